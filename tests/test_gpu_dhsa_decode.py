"""DHSA decode on the GPU against the CPU oracle: the new query sits in the
current, partial chunk; complete chunks are scored through the pooled-key
cache built by dhsa_build_chunk_keys."""
import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import oracle
import synth
from gpu_util import MARGIN, check_exempt, check_out, dev, gen, host, say

pytestmark = pytest.mark.gpu


def check_order(order, sc, what):
    """The GPU's chunk ranking against the oracle's S_c: wherever adjacent
    oracle scores differ by more than the margin, the ranking must agree."""
    B, H, nc = sc.shape
    for b in range(B):
        for h in range(H):
            s = sc[b, h]
            ref = np.lexsort((np.arange(nc), -s))
            got = order[b, h]
            assert sorted(got.tolist()) == list(range(nc)), what
            # positions where the reference's neighbours are well separated
            gaps = -np.diff(s[ref])
            for p in range(nc):
                lo_ok = p == 0 or gaps[p - 1] > MARGIN
                hi_ok = p == nc - 1 or gaps[p] > MARGIN
                if lo_ok and hi_ok:
                    assert got[p] == ref[p], f"{what}: b={b} h={h} rank {p}"


def run_case(B, H, d, dt, offs_all, n, m, budget, seed, n_max=None):
    """Decode of the query at offs_all[n] + m - 1 with complete chunks 0..n-1."""
    offs = np.asarray(offs_all[: n + 1], np.int32)
    pos = int(offs[-1]) + m - 1
    n_max = n_max or pos + 1
    say(f"dhsa decode B={B} H={H} d={d} {dt} n={n} m={m} pos={pos} budget={budget}")
    Q = gen((B, H, n_max, d), dt, seed, synth.TID_Q)
    K = gen((B, H, n_max, d), dt, seed, synth.TID_K)
    V = gen((B, H, n_max, d), dt, seed, synth.TID_V)
    qcur = np.ascontiguousarray(Q[:, :, offs[-1]: pos + 1])
    kd, vd = dev(K), dev(V)
    khat = hsa.dhsa_build_chunk_keys(kd, offs, n_cap=n + 3)
    o, order = hsa.dhsa_decode(dev(qcur), kd, vd, khat, offs, budget, return_order=True)
    torch.cuda.synchronize()
    o, order = host(o), host(order)
    ref = oracle.dhsa_decode(qcur, K, V, offs, budget)
    check_order(order, ref["sc"], "chunk order")
    ok = ref["margin"] > MARGIN
    check_exempt(ok, "dhsa decode rows")
    err = check_out(o[ok], ref["out"][ok], dt, "dhsa decode output") if ok.any() else 0.0
    say(f"  ok: max err {err:.3g}, exempt {1 - ok.mean():.3f}")
    return khat, K, offs


SWEEP = [
    # B, H, d, dtype, chunk lengths lo..hi, n complete, m, budget
    (2, 3, 128, "bf16", 16, 128, 20, 7, 300),
    (1, 2, 64, "f32", 4, 40, 30, 1, 50),
    (1, 4, 128, "bf16", 16, 128, 60, 128, 2048),
    (3, 1, 64, "bf16", 1, 1, 70, 1, 9),        # unit chunks
    (1, 2, 128, "f32", 10, 30, 12, 25, 10 ** 6),  # budget covers everything
    (1, 2, 128, "bf16", 200, 700, 9, 300, 1500),  # chunks longer than 256 keys
    (2, 2, 64, "bf16", 5, 9, 0, 6, 4),          # no complete chunk yet
    (1, 1, 128, "bf16", 5, 9, 0, 1, 1),         # the very first token
    # the chunk ranking counts larger keys up to 1024 chunks (+ the current
    # one) and sorts bitonically beyond: both sides of the switch
    (1, 2, 64, "bf16", 1, 1, 1023, 1, 700),
    (1, 2, 64, "bf16", 1, 1, 1500, 1, 700),
]


@pytest.mark.parametrize("case", SWEEP, ids=[str(i) for i in range(len(SWEEP))])
def test_dhsa_decode_sweep(case):
    B, H, d, dt, lo, hi, n, m, budget = case
    seed = 40 + SWEEP.index(case)
    offs_all = synth.chunk_offsets(max(n, 1) * hi + 4 * hi, lo, hi, seed=seed)
    assert len(offs_all) > n
    run_case(B, H, d, dt, offs_all, n, m, budget, seed)


def test_chunk_keys_match_oracle_and_append():
    B, H, d = 2, 3, 128
    offs = synth.chunk_offsets(3000, 16, 128, seed=48)
    n = len(offs) - 1
    K = gen((B, H, 3000, d), "bf16", 48, synth.TID_K)
    kd = dev(K)
    full = hsa.dhsa_build_chunk_keys(kd, offs)
    torch.cuda.synchronize()
    ref = oracle.dhsa_chunk_keys(K, offs)
    np.testing.assert_allclose(host(full), ref, rtol=2e-6, atol=2e-6)
    # growing the cache chunk by chunk gives the same rows
    part = torch.zeros_like(full)
    hsa.dhsa_build_chunk_keys(kd, offs[: n - 3], khat=part)  # chunks 0 .. n-5
    for k in range(n - 4, n):
        hsa.dhsa_build_chunk_keys(kd, offs[: k + 2], chunk_begin=k, chunk_end=k + 1, khat=part)
    torch.cuda.synchronize()
    assert torch.equal(part, full)


def test_decode_equals_prefill_row_on_the_gpu():
    # the decode step equals dhsa_prefill's last row of the sequence cut at
    # the new token, on the same device
    B, H, d, budget = 1, 4, 128, 700
    offs_all = synth.chunk_offsets(4096, 16, 128, seed=49)
    n = len(offs_all) - 2
    m = 11
    pos = int(offs_all[n]) + m - 1
    Q = gen((B, H, pos + 1, d), "bf16", 49, synth.TID_Q)
    K = gen((B, H, pos + 1, d), "bf16", 49, synth.TID_K)
    V = gen((B, H, pos + 1, d), "bf16", 49, synth.TID_V)
    offs = offs_all[: n + 1]
    qd, kd, vd = dev(Q), dev(K), dev(V)
    khat = hsa.dhsa_build_chunk_keys(kd, offs)
    dec = hsa.dhsa_decode(qd[:, :, offs[-1]:].contiguous(), kd, vd, khat, offs, budget)
    pre = hsa.dhsa_prefill(qd, kd, vd, np.append(offs, pos + 1), budget)
    torch.cuda.synchronize()
    diff = np.abs(host(dec) - host(pre)[:, :, pos]).max()
    assert diff <= 1e-2, diff


def test_dhsa_decode_16k_context():
    # the 16K-token DHSA sequence decoding its last token (its last chunk is
    # the current one), batch 4, 8 heads, N_b = 2048
    B, H, d, budget = 4, 8, 128, 2048
    offs_all = synth.chunk_offsets(16384, 16, 128, seed=5)
    n = len(offs_all) - 2
    m = int(offs_all[-1] - offs_all[-2])
    run_case(B, H, d, "bf16", offs_all, n, m, budget, seed=50)
