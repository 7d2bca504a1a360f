"""hsa_decode_noalloc (the decode entry point that uses the library's fixed
device scratch instead of a caller workspace) against hsa_decode: two calls
in a row, the second on a smaller input, each bit for bit equal to
hsa_decode's output and selection and within the oracle's bar; and a shape
above the scratch size is rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import oracle
import synth
from gpu_util import MARGIN, check_out, dev, gen, host, say

pytestmark = pytest.mark.gpu


def one_call(B, Hq, Hkv, n_max, n_ctx, d, S, K, dt, seed):
    say(f"noalloc decode B={B} Hq={Hq} Hkv={Hkv} n_ctx={n_ctx} S={S} K={K} {dt}")
    q = gen((B, Hq, d), dt, seed, synth.TID_QDEC)
    Kc = gen((B, Hkv, n_max, d), dt, seed, synth.TID_K)
    Vc = gen((B, Hkv, n_max, d), dt, seed, synth.TID_V)
    lmk = np.zeros((B, Hkv, n_max // S, d), np.float32)
    n = n_ctx // S
    lmk[:, :, :n] = oracle.landmarks(Kc[:, :, : n * S], S).astype(np.float32)
    qd, kd, vd, ld = dev(q), dev(Kc), dev(Vc), dev(lmk)
    ref_o, ref_sel, ref_w = hsa.hsa_decode(qd, kd, vd, ld, n_ctx, S, K, return_selection=True)
    out = torch.empty_like(qd)
    sel = torch.empty((B, Hkv, K), dtype=torch.int32, device=qd.device)
    w = torch.empty((B, Hq, K), dtype=torch.float32, device=qd.device)
    hsa.hsa_decode_noalloc(qd, kd, vd, ld, n_ctx, S, K, out, sel, w)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if dt == "bf16" else out,
                       ref_o.view(torch.int16) if dt == "bf16" else ref_o), "output differs"
    assert torch.equal(sel, ref_sel), "selection differs"
    assert torch.equal(w, ref_w), "fusion weights differ"
    r = oracle.hsa_decode(q, Kc, Vc, lmk, S, n_ctx, K)
    ok = (r["margin"] > MARGIN).all(-1)
    err = check_out(host(out)[ok], r["out"][ok], dt, "noalloc decode output")
    say(f"  ok: max err {err:.3g}, rows checked {int(ok.sum())} of {ok.size}")


def test_noalloc_decode_matches_decode_two_calls():
    one_call(4, 16, 4, 12000, 11000, 128, 64, 8, "bf16", seed=401)
    # a smaller input second: the scratch still holds the first call's data
    one_call(2, 8, 2, 3000, 2999, 64, 32, 4, "f32", seed=402)


def test_noalloc_rejects_shapes_above_the_scratch():
    lib = hsa.load_library()
    need = lib.hsa_decode_workspace_size(64, 64, 8, 128, 64, 32, 1 << 20)
    assert need > hsa.HSA_DECODE_NOALLOC_SCRATCH_BYTES
    rc = lib.hsa_decode_noalloc(None, None, None, None, 1 << 20, 1 << 20, None, None, None, 64,
                                64, 8, 128, 64, 32, hsa.DTYPE_BF16, None)
    assert rc == hsa.HSA_ERR_UNSUPPORTED
    assert "scratch" in lib.hsa_last_error_message().decode()


def test_noalloc_decode_replays_under_graph_capture():
    # The callers this entry point is for run it under HIP graph capture:
    # capture one call, then replay it several times with eager calls in
    # between, one of them on another shape (it rewrites the shared scratch
    # with its own data); every replay equals the eager hsa_decode bit for bit
    say("noalloc decode captured in a HIP graph, 4 replays")
    B, Hq, Hkv, n_max, n_ctx, d, S, K = 4, 16, 4, 12000, 11000, 128, 64, 8
    q = gen((B, Hq, d), "bf16", 403, synth.TID_QDEC)
    Kc = gen((B, Hkv, n_max, d), "bf16", 403, synth.TID_K)
    Vc = gen((B, Hkv, n_max, d), "bf16", 403, synth.TID_V)
    lmk = np.zeros((B, Hkv, n_max // S, d), np.float32)
    lmk[:, :, : n_ctx // S] = oracle.landmarks(Kc[:, :, : n_ctx // S * S], S).astype(np.float32)
    qd, kd, vd, ld = dev(q), dev(Kc), dev(Vc), dev(lmk)
    ref_o, ref_sel, ref_w = hsa.hsa_decode(qd, kd, vd, ld, n_ctx, S, K, return_selection=True)
    out = torch.empty_like(qd)
    sel = torch.empty((B, Hkv, K), dtype=torch.int32, device=qd.device)
    w = torch.empty((B, Hq, K), dtype=torch.float32, device=qd.device)
    # the other shape's inputs (fp32, d = 64, S = 32, top-4)
    q2 = gen((2, 8, 64), "f32", 404, synth.TID_QDEC)
    K2 = gen((2, 2, 3000, 64), "f32", 404, synth.TID_K)
    V2 = gen((2, 2, 3000, 64), "f32", 404, synth.TID_V)
    l2 = np.zeros((2, 2, 3000 // 32, 64), np.float32)
    l2[:, :, : 2999 // 32] = oracle.landmarks(K2[:, :, : 2999 // 32 * 32], 32).astype(np.float32)
    q2d, k2d, v2d, l2d = dev(q2), dev(K2), dev(V2), dev(l2)
    ref2 = hsa.hsa_decode(q2d, k2d, v2d, l2d, 2999, 32, 4)
    out2 = torch.empty_like(q2d)
    # warm-up on a side stream (the first call looks up the scratch address)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        hsa.hsa_decode_noalloc(qd, kd, vd, ld, n_ctx, S, K, out, sel, w)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        hsa.hsa_decode_noalloc(qd, kd, vd, ld, n_ctx, S, K, out, sel, w)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        sel.fill_(-7)
        w.zero_()
        if rep % 2:
            hsa.hsa_decode_noalloc(q2d, k2d, v2d, l2d, 2999, 32, 4, out2)
            torch.cuda.synchronize()
            assert torch.equal(out2, ref2), "eager call between replays differs"
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep}: output"
        assert torch.equal(sel, ref_sel), f"replay {rep}: selection"
        assert torch.equal(w, ref_w), f"replay {rep}: fusion weights"
    say("  ok: 4 replays equal the eager call")
