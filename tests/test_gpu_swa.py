"""Sliding-window attention (the local attention of the upper layers) on the
GPU against the CPU oracle: prefill over whole sequences, decode of one new
token, and a decode loop that appends keys, values and landmarks as it goes
(the memory update beside the HSA decode)."""
import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import oracle
import synth
from gpu_util import by_chunk, check_out, compare_selection, dev, gen, host, qkv, say

pytestmark = pytest.mark.gpu


def run_prefill(B, Hq, Hkv, L, d, W, dt, seed, rows=None, scale=1.0):
    say(f"swa prefill B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} W={W} {dt}")
    Q, K, V = qkv(B, Hq, Hkv, L, d, dt, seed, scale)
    out = hsa.swa_prefill(dev(Q), dev(K), dev(V), W)
    torch.cuda.synchronize()
    out = host(out)
    ref = oracle.swa_prefill(Q, K, V, W, rows=rows)
    got = out if rows is None else out[:, :, rows]
    err = check_out(got, ref, dt, "swa prefill output")
    say(f"  ok: max err {err:.3g}")


PREFILL = [
    # B, Hq, Hkv, L, d, W, dtype
    (1, 16, 4, 2000, 128, 512, "bf16"),  # the upper-layer window, ragged tail
    (2, 8, 8, 777, 64, 100, "bf16"),     # no grouping: 128 positions per block
    (1, 8, 4, 300, 128, 1, "bf16"),      # a window of one: the own value
    (1, 4, 2, 700, 128, 5000, "bf16"),   # window past the sequence: dense causal
    (1, 6, 2, 513, 128, 33, "bf16"),     # groups of 3 heads
    (1, 16, 2, 600, 128, 512, "bf16"),   # groups of 8 heads: two head blocks
    (2, 4, 2, 400, 128, 64, "f32"),
    (1, 4, 1, 300, 64, 200, "f32"),
    (1, 2, 1, 1, 128, 512, "bf16"),      # a single token
]


@pytest.mark.parametrize("case", PREFILL, ids=[str(i) for i in range(len(PREFILL))])
def test_swa_prefill_sweep(case):
    run_prefill(*case, seed=200 + PREFILL.index(case))


def test_swa_prefill_32k_workload():
    # the 32K GQA bf16 sequence of the upper layers, 512-token window:
    # sampled rows (window edges, tile edges, the end)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.integers(0, 32768, 300), np.arange(0, 32768, 4099),
                                     [0, 1, 31, 32, 510, 511, 512, 513, 32736, 32767]]))
    run_prefill(1, 16, 4, 32768, 128, 512, "bf16", seed=12, rows=rows, scale=0.5)


def run_decode(B, Hq, Hkv, n_max, pos, d, W, dt, seed):
    say(f"swa decode B={B} Hq={Hq} Hkv={Hkv} n_max={n_max} pos={pos} d={d} W={W} {dt}")
    q = gen((B, Hq, d), dt, seed, synth.TID_QDEC)
    K = gen((B, Hkv, n_max, d), dt, seed, synth.TID_K)
    V = gen((B, Hkv, n_max, d), dt, seed, synth.TID_V)
    o = hsa.swa_decode(dev(q), dev(K), dev(V), pos, W)
    torch.cuda.synchronize()
    ref = oracle.swa_decode(q, K, V, pos, W)
    err = check_out(host(o), ref, dt, "swa decode output")
    say(f"  ok: max err {err:.3g}")


DECODE = [
    # B, Hq, Hkv, n_max, pos, d, W, dtype
    (4, 32, 8, 3000, 2999, 128, 512, "bf16"),
    (2, 8, 2, 1000, 5, 128, 512, "bf16"),     # fewer tokens than the window
    (3, 4, 4, 700, 650, 64, 100, "f32"),
    (1, 6, 2, 5000, 4321, 128, 1000, "bf16"),  # several pieces per wave
    (1, 4, 2, 100, 0, 128, 512, "bf16"),      # the first token
    (2, 8, 4, 300, 299, 128, 1, "bf16"),      # a window of one
    (2, 16, 2, 2048, 1500, 128, 512, "f32"),
]


@pytest.mark.parametrize("case", DECODE, ids=[str(i) for i in range(len(DECODE))])
def test_swa_decode_sweep(case):
    run_decode(*case, seed=220 + DECODE.index(case))


def test_swa_decode_equals_prefill_row_on_the_gpu():
    B, Hq, Hkv, L, d, W = 2, 16, 4, 1500, 128, 512
    Q, K, V = qkv(B, Hq, Hkv, L, d, "bf16", 230)
    qd, kd, vd = dev(Q), dev(K), dev(V)
    pre = hsa.swa_prefill(qd, kd, vd, W)
    for pos in (0, 100, 511, 512, 1499):
        dec = hsa.swa_decode(qd[:, :, pos].contiguous(), kd, vd, pos, W)
        torch.cuda.synchronize()
        diff = float((dec.float() - pre[:, :, pos].float()).abs().max())
        assert diff <= 1e-2, (pos, diff)


def test_swa_decode_batch32_131k_cache():
    # batch 32 decoding at the end of 131072-token caches (32 over 8 heads):
    # the caches come from the device generator; the host regenerates only
    # the window
    B, Hq, Hkv, N, d, W, seed = 32, 32, 8, 131072, 128, 512, 9
    say("swa decode batch 32, 131072-token caches")
    Kc = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device="cuda")
    Vc = torch.empty_like(Kc)
    synth.normal_device(Kc, seed, synth.TID_K)
    synth.normal_device(Vc, seed, synth.TID_V)
    q = synth.normal((B, Hq, d), synth.BF16, seed, synth.TID_QDEC)
    pos = N - 1
    o = host(hsa.swa_decode(dev(q), Kc, Vc, pos, W))
    torch.cuda.synchronize()
    Kw = np.empty((B, Hkv, W, d), np.uint16)
    Vw = np.empty_like(Kw)
    for b in range(B):
        for g in range(Hkv):
            first = ((b * Hkv + g) * N + pos - W + 1) * d
            Kw[b, g] = synth.normal((W, d), synth.BF16, seed, synth.TID_K, first=first)
            Vw[b, g] = synth.normal((W, d), synth.BF16, seed, synth.TID_V, first=first)
    # the device caches hold the same window
    assert np.array_equal(Kc[3, 5, pos - W + 1:pos + 1].view(torch.int16).cpu().numpy().view(
        np.uint16), Kw[3, 5])
    ref = oracle.swa_decode(q, Kw, Vw, W - 1, W)
    err = check_out(o, ref, "bf16", "swa decode 131k")
    say(f"  ok: max err {err:.3g}")
    del Kc, Vc
    torch.cuda.empty_cache()


def test_upper_layer_decode_loop_with_landmark_append():
    # token by token: append k, v to the caches, append the landmark of each
    # chunk the moment it completes, then the sliding-window and the HSA
    # decode of the new query; both against the oracle on the full sequence
    B, Hq, Hkv, d, S, topk, W, n_max = 1, 8, 2, 128, 16, 4, 40, 200
    seed = 240
    Q, K, V = qkv(B, Hq, Hkv, n_max, d, "bf16", seed)
    Kc = torch.zeros((B, Hkv, n_max, d), dtype=torch.bfloat16, device="cuda")
    Vc = torch.zeros_like(Kc)
    lmk = torch.zeros((B, Hkv, n_max // S, d), dtype=torch.float32, device="cuda")
    kd, vd, qd = dev(K), dev(V), dev(Q)
    steps = list(range(0, 120)) + [150, 199]
    ref_swa = oracle.swa_prefill(Q, K, V, W, rows=steps)
    ref_hsa = oracle.hsa_prefill(Q, K, V, S, topk, rows=steps)
    t_done = 0
    for r, t in enumerate(steps):
        # cache and memory update up to and including token t
        Kc[:, :, t_done:t + 1] = kd[:, :, t_done:t + 1]
        Vc[:, :, t_done:t + 1] = vd[:, :, t_done:t + 1]
        c0, c1 = t_done // S, (t + 1) // S
        if c1 > c0:
            hsa.hsa_build_landmarks(Kc, S, chunk_begin=c0, chunk_end=c1, lmk=lmk)
        t_done = t + 1
        q = qd[:, :, t].contiguous()
        o_swa = hsa.swa_decode(q, Kc, Vc, t, W)
        o_hsa, sel, w = hsa.hsa_decode(q, Kc, Vc, lmk, t, S, topk, return_selection=True)
        torch.cuda.synchronize()
        check_out(host(o_swa), ref_swa[:, :, r], "bf16", f"swa decode at {t}")
        sel_ref = ref_hsa["sel"][:, :, r]
        same, _ = compare_selection(host(sel)[:, :, None], sel_ref[:, :, None],
                                    ref_hsa["margin"][:, :, r:r + 1], f"hsa selection at {t}")
        ok = np.repeat(same[:, :, 0], Hq // Hkv, axis=1)
        check_out(host(o_hsa)[ok], ref_hsa["out"][:, :, r][ok], "bf16", f"hsa decode at {t}")
    say(f"  ok: {len(steps)} decode steps")
