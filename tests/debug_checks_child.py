"""Runs every compute entry point once on seeded inputs and saves the outputs
to the .npz named on the command line.  tests/test_gpu_debug_checks.py runs
it twice, with HSA_ATTN_DEBUG=1 (the device-checked library, which turns any
failed check into an error) and with HSA_ATTN_DEBUG=0, and compares."""
import sys

import numpy as np
import torch

import chunk_hierarchical_sparse_amd as hsa
import synth
from gpu_util import dev, gen, host, qkv


def main(path):
    print("library:", hsa.lib_path(), "checks:", hsa.hsa_device_checks_enabled(), flush=True)
    res = {}
    if hsa.hsa_device_checks_enabled():
        # the self-test: a passing check, a failing one (reported, then
        # cleared), and a passing one again
        lib = hsa.load_library()
        s0 = hsa.hsa_device_checks_selftest(False)
        s1 = hsa.hsa_device_checks_selftest(True)
        res["selftest_msg"] = np.array(lib.hsa_last_error_message().decode())
        s2 = hsa.hsa_device_checks_selftest(False)
        hsa.hsa_device_checks_selftest(True)
        res["selftest_msg2"] = np.array(lib.hsa_last_error_message().decode())
        res["selftest"] = np.array([s0, s1, s2])
    B, Hq, Hkv, L, d, S, K = 1, 8, 2, 4096, 128, 64, 8
    Q, Kx, V = qkv(B, Hq, Hkv, L, d, "bf16", 7, 0.5)
    q, k, v = dev(Q), dev(Kx), dev(V)
    print("hsa_prefill", flush=True)
    o, sel, w = hsa.hsa_prefill(q, k, v, S, K, return_selection=True)
    res.update(prefill_o=host(o), prefill_sel=host(sel), prefill_w=host(w))
    print("hsa_prefill_interval", flush=True)
    o, sel, _ = hsa.hsa_prefill_interval(q, k, v, S, K, 8, return_selection=True)
    res.update(interval_o=host(o), interval_sel=host(sel))
    print("hsa_prefill_backward", flush=True)
    dO = dev(gen((B, Hq, L, d), "bf16", 7, synth.TID_DO))
    dq, dk, dv = hsa.hsa_prefill_backward(q, k, v, dO, S, K)
    res.update(bwd_dq=host(dq), bwd_dk=host(dk), bwd_dv=host(dv))
    print("hsa_swa_prefill", flush=True)
    oh, osw = hsa.hsa_swa_prefill(q, k, v, S, K, 512)
    res.update(upper_hsa=host(oh), upper_swa=host(osw))
    print("swa_prefill", flush=True)
    res["swa_prefill"] = host(hsa.swa_prefill(q, k, v, 300))
    print("hsa_decode", flush=True)
    lmk = hsa.hsa_build_landmarks(k, S)
    res["lmk"] = host(lmk)
    qd = q[:, :, L - 1].contiguous()
    o, sel, _ = hsa.hsa_decode(qd, k, v, lmk, L - 1, S, K, return_selection=True)
    res.update(decode_o=host(o), decode_sel=host(sel))
    print("hsa_swa_decode", flush=True)
    oh, osw = hsa.hsa_swa_decode(qd, k, v, lmk, L - 1, S, K, 700)
    res.update(swa_decode_hsa=host(oh), swa_decode_swa=host(osw))
    print("swa_decode", flush=True)
    res["swa_decode"] = host(hsa.swa_decode(qd, k, v, L - 1, 700))
    for dt in ("bf16", "f32"):
        print("dhsa_prefill", dt, flush=True)
        Ld, H = 2000, 2
        offs = synth.chunk_offsets(Ld, 16, 128, seed=11)
        Qd, Kd, Vd = qkv(1, H, H, Ld, d, dt, 11)
        o, mask, order = hsa.dhsa_prefill(dev(Qd), dev(Kd), dev(Vd), offs, 300, return_mask=True,
                                          return_order=True)
        res.update({f"dhsa_o_{dt}": host(o), f"dhsa_mask_{dt}": host(mask),
                    f"dhsa_order_{dt}": host(order)})
        print("dhsa_decode", dt, flush=True)
        n = len(offs) - 3
        pos = int(offs[n]) + 5
        qcur = dev(np.ascontiguousarray(Qd[:, :, offs[n]: pos + 1]))
        kd = dev(Kd)
        khat = hsa.dhsa_build_chunk_keys(kd, offs[: n + 1], n_cap=n + 2)
        o, order = hsa.dhsa_decode(qcur, kd, dev(Vd), khat, offs[: n + 1], 300,
                                   return_order=True)
        res.update({f"dhsa_dec_o_{dt}": host(o), f"dhsa_dec_order_{dt}": host(order),
                    f"khat_{dt}": host(khat)})
    torch.cuda.synchronize()
    np.savez(path, **res)
    print("saved", path, flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
