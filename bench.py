#!/usr/bin/env python3
"""Throughput of the hierarchical sparse attention forward path on one MI355X.

One step = one call of the whole path on one batch of synthetic input that is
already resident in HBM.  The headline workload is HSA prefill at B=1,
L=32768, 16 query heads over 4 KV heads, d=128, S=64, top-8, bf16: landmark
pooling, scoring + top-K, chunk attention and fusion, all inside the timed
call.  By default the decode workloads (batch 32 with 131072-token caches;
batch 1 with a 16,777,216-token cache and a planted needle), the DHSA
prefill workload (L=16384, N_b=2048), DHSA decode (that sequence decoding
its last token, batch 32), the 32K prefill with retrieval every 8 tokens and
the sliding-window attention of the upper layers (512-token window, over the
32K prefill inputs and at the end of the batch-32 decode caches) and the
prefill backward (gradients of the 32K prefill for an N(0,1) output
gradient) are measured too and reported under "also".

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
METRIC = "HSA queries/sec + achieved HBM GB/s (decode) / MFMA util (prefill), 1 GPU"

# The dominant kernel of each workload (a substring of its demangled name and
# its argument struct) and the sources it is built from.  HBM traffic per
# launch comes from rocprofv3 FETCH_SIZE / WRITE_SIZE runs summarised by
# --summarize-counters into TRAFFIC_FILE; it is reported only while these
# sources hash the same as when the counters were taken.
CSRC = os.path.join(ROOT, "chunk_hierarchical_sparse_amd", "csrc")
PREFILL_SRC = ["prefill.hip", "chunk_attend.h", "prefill_common.h", "attn_core.h", "hsa_common.h",
               "kernels.h"]
DOMINANT = {
    "hsa_prefill": ("attend_chunk_bf16_kernel<128, true>", "PrefillArgs", PREFILL_SRC),
    "hsa_prefill_r8": ("qmajor_kernel<128>", "PrefillArgs",
                       ["prefill_qmajor.hip", "attn_core.h", "hsa_common.h", "kernels.h"]),
    "hsa_decode": ("scan_kernel<128, 1>", "DecodeArgs",
                   ["decode.hip", "hsa_common.h", "kernels.h"]),
    "hsa_decode_16m": ("scan_kernel<128, 1>", "DecodeArgs",
                       ["decode.hip", "hsa_common.h", "kernels.h"]),
    "dhsa_prefill": ("attend_kernel<128, 4>", "DhsaArgs",
                     ["dhsa.hip", "attn_core.h", "hsa_common.h", "kernels.h"]),
    "dhsa_decode": ("attend_kernel<128, 1>", "DhsaDecodeArgs",
                    ["dhsa_decode.hip", "hsa_common.h", "kernels.h"]),
    "hsa_prefill_backward": ("bwd_kv_kernel<128>", "PrefillBwdArgs",
                             ["prefill_bwd.hip", "prefill_common.h", "attn_core.h",
                              "hsa_common.h", "kernels.h"]),
    "swa_prefill": ("prefill_bf16_kernel<128, 4>", "SwaArgs",
                    ["swa.hip", "swa_core.h", "attn_core.h", "hsa_common.h", "kernels.h"]),
    "swa_decode": ("decode_kernel<128, 1, 4>", "SwaArgs",
                   ["swa.hip", "hsa_common.h", "kernels.h"]),
    "hsa_swa_prefill": ("upper_attend_kernel<128, true, 4>", "PrefillArgs",
                        ["upper.hip", "chunk_attend.h", "swa_core.h", "prefill_common.h",
                         "attn_core.h", "hsa_common.h", "kernels.h"]),
}
# Other kernels whose HBM traffic the counter summary records per workload
# (name, argument struct, sources): the prefill fusion, for the traffic floor
# of the chunk-major schedule.
SECONDARY = {
    "hsa_prefill": ("fuse_kernel<128, 1, 8>", "PrefillArgs", PREFILL_SRC),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_bench_workloads.txt")


SQ_FILE = os.path.join(ROOT, "profiles", "sq_counters_bench_workloads.txt")


def sources_sha1(workload, table=None):
    import hashlib
    h = hashlib.sha1()
    for f in (table or DOMINANT)[workload][2]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _profile_record(path, key, workload):
    """The record of `workload` under `key` in a committed profile summary
    (JSON after '#' comment lines), or None when absent or taken on other
    sources."""
    try:
        with open(path) as fh:
            body = "".join(l for l in fh if not l.lstrip().startswith("#"))
        rec = json.loads(body)[key][workload]
    except (OSError, ValueError, KeyError, TypeError):
        return None
    return rec if rec.get("sources_sha1") == sources_sha1(workload) else None


def mfma_busy_for(workload):
    """MFMA-busy and VALU-busy percentages and executed / algorithmic MFMA
    flops of the workload's dominant kernel from the SQ counter summary, or
    None when absent or taken on other sources."""
    rec = _profile_record(SQ_FILE, "workloads", workload)
    if rec is None:
        return None
    return {k: rec[k] for k in ("mfma_busy_pct", "valu_busy_pct", "executed_over_algorithmic")}


def traffic_for(workload):
    """HBM bytes per launch of the workload's dominant kernel from the
    counter summary, or None when absent or taken on other sources."""
    rec = _profile_record(TRAFFIC_FILE, "workloads", workload)
    return None if rec is None else rec["traffic_bytes"]


def secondary_traffic_for(workload):
    """HBM bytes per launch of the workload's secondary kernel (SECONDARY),
    or None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            body = "".join(l for l in fh if not l.lstrip().startswith("#"))
        rec = json.loads(body)["secondary"][workload]
    except (OSError, ValueError, KeyError, TypeError):
        return None
    if rec.get("sources_sha1") != sources_sha1(workload, SECONDARY):
        return None
    return rec["traffic_bytes"]


def hbm_view(traffic, ms):
    """The kernel's counter-measured HBM bytes per launch over its measured
    duration, against the HBM peak: how close the schedule's own traffic
    runs to the memory roofline (null without counter data)."""
    if traffic is None or not ms:
        return None
    gbps = traffic / (ms * 1e-3) / 1e9
    return {"bytes_per_launch": traffic, "achieved": gbps, "unit": "GB/s",
            "peak": PEAK_HBM_GBPS, "frac": gbps / PEAK_HBM_GBPS}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(arr, torch):
    import numpy as np
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(
            torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


class Flush:
    """Cache flush run before every timed call, outside its events, so that no
    call finds data the previous one left in the L2 or the 256 MB Infinity
    Cache.  It writes a 1 GiB scratch buffer; in the default "write-read"
    mode it then reads the buffer back.  A write alone leaves the last
    ~288 MB it wrote dirty in the caches, and the timed call then pays for
    writing them back to HBM as its own reads evict them (a probe of the
    sliding-window decode's reads: 31-34 us after a write, 15-19 us after a
    write followed by a read).  The read-back evicts them (written back
    outside the events) and leaves clean lines of the scratch buffer, so the
    timed call starts from cold, clean caches.  "write" keeps the write only."""

    def __init__(self, torch, gib=1.0, mode="write-read"):
        self.buf = torch.empty(int(gib * (1 << 30)), dtype=torch.uint8, device="cuda")
        self.words = self.buf.view(torch.int64)
        self.mode = mode
        self.k = 0

    def __call__(self):
        self.k ^= 1
        self.buf.fill_(self.k)
        if self.mode == "write-read":
            self.words.max()  # reads every byte back; the result is not used

    def describe(self):
        return ("a 1 GiB cache-flush write, then a read of it" if self.mode == "write-read"
                else "a 1 GiB cache-flush write")


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return 0.0 if n == 0 else (xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2]))


def time_steps(torch, hsa, step, steps, warmup, n_stages, flush):
    """Warm-up calls, then `steps` timed calls, each after a cache flush and
    between its own pair of HIP events on the library's stream (torch's
    current stream): the step time is their median.  Then `steps` more
    calls, again each after a flush, with the library's per-stage HIP events
    on: the events between the kernels cost a few microseconds each, so they
    stay out of the step time.  Every workload therefore launches its
    kernels warmup + 2 * steps times.

    Returns dict(ms = median step, ms_mean, stage_mean = per-stage mean ms,
    stage_median = per-stage median ms)."""
    for _ in range(warmup):
        flush()
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        flush()
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in ev]
    hsa.hsa_profile_read()  # drop anything recorded earlier
    per_call = []
    for _ in range(steps):
        flush()
        hsa.hsa_profile_enable(True)
        step()
        hsa.hsa_profile_enable(False)
        calls, st = hsa.hsa_profile_read(n_stages)
        per_call.append(st if calls == 1 else [0.0] * n_stages)
    torch.cuda.synchronize()
    cols = list(zip(*per_call)) if per_call else [()] * n_stages
    return {"ms": _median(times), "ms_mean": sum(times) / len(times),
            "stage_mean": [sum(c) / max(len(c), 1) for c in cols],
            "stage_median": [_median(list(c)) for c in cols]}


def add_timing(res, t, stage):
    """Adds the mean step time and the dominant kernel's median launch time
    (stage `stage`) beside the median step time and mean launch time the
    record already holds, and for MFMA-bound kernels the SQ counters'
    MFMA-busy corroboration."""
    res["ms_per_step_mean"] = t["ms_mean"]
    res["roofline"]["median_launch_ms"] = t["stage_median"][stage]
    if res["roofline"]["bound"] == "mfma":
        res["roofline"]["mfma_busy"] = mfma_busy_for(res["config"]["workload"])
    return res


def measure_copy_rate(torch, flush, reps=5):
    """Bytes moved per second (read + write) by a plain 1 GiB device copy,
    median of `reps`, each after a cache flush: the rate the traffic floor is
    priced at."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ts = []
    for _ in range(reps):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n / (_median(ts) * 1e-3)


def prefill_counts(L, S, topk):
    """Per (b, group): selected (token, chunk) pairs and available chunks."""
    n = L // S
    sel = avail = 0
    for t in range(L):
        a = min(t // S, n)
        avail += a
        sel += min(topk, a)
    return sel, avail


def prefill_traffic_floor(copy_rate, attend_fuse_ms):
    """The chunk-major schedule's traffic floor: the HBM bytes its attention
    and fusion kernels move per call (counter summary) priced at the plain
    copy rate measured in this run, beside their measured time."""
    ta, tf = traffic_for("hsa_prefill"), secondary_traffic_for("hsa_prefill")
    if ta is None or tf is None:
        return None
    return {"attend_bytes": ta, "fuse_bytes": tf, "copy_GBps": copy_rate / 1e9,
            "floor_ms": (ta + tf) / copy_rate * 1e3, "attend_plus_fuse_ms": attend_fuse_ms}


# ---------------------------------------------------------------- workloads


def bench_prefill(torch, hsa, args):
    import synth
    B, Hq, Hkv, L, d, S, topk = 1, 16, 4, 32768, 128, 64, 8
    log("prefill: generating inputs")
    Q = synth.normal((B, Hq, L, d), synth.BF16, 2, synth.TID_Q, 0.5)
    K = synth.normal((B, Hkv, L, d), synth.BF16, 2, synth.TID_K, 0.5)
    V = synth.normal((B, Hkv, L, d), synth.BF16, 2, synth.TID_V, 0.5)
    q, k, v = to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch)
    out = torch.empty_like(q)
    ws = torch.empty(hsa.hsa_prefill_workspace_size(B, L, Hq, Hkv, d, S, topk, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def step():
        hsa.hsa_prefill(q, k, v, S, topk, out=out, workspace=ws)

    log("prefill: timing")
    t = time_steps(torch, hsa, step, args.steps, args.warmup, 5, args.flush)
    ms, stages = t["ms"], t["stage_mean"]
    sel, avail = prefill_counts(L, S, topk)
    attn_flop = B * Hq * sel * S * d * 4          # QK^T + PV over selected chunks
    score_flop = B * Hkv * avail * d * 2          # group-summed retrieval scores
    fuse_flop = B * Hq * sel * d * 2              # per-head scores of kept chunks
    total_flop = attn_flop + score_flop + fuse_flop
    attn_ms = stages[3]
    achieved = attn_flop / (attn_ms * 1e-3) / 1e12
    res = dict(
        value=B * L / (ms * 1e-3), ms_per_step=ms,
        config={"workload": "hsa_prefill", "B": B, "L": L, "Hq": Hq, "Hkv": Hkv, "d": d,
                "S": S, "topk": topk, "inputs": "0.5*N(0,1) bf16, seed 2"},
        roofline={"bound": "mfma", "kernel": "attend (chunk attention, bf16 MFMA)",
                  "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                  "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic_for("hsa_prefill"),
                  "algorithmic_gflop_per_launch": attn_flop / 1e9, "avg_launch_ms": attn_ms,
                  "hbm_view": hbm_view(traffic_for("hsa_prefill"), attn_ms)},
        stages_ms=dict(zip(["landmarks", "select", "invert", "attend", "fuse"], stages)),
        traffic_floor=prefill_traffic_floor(args.copy_rate, stages[3] + stages[4]),
        whole_path={"gflop": total_flop / 1e9,
                    "tflops": total_flop / (ms * 1e-3) / 1e12,
                    "mfma_frac": total_flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS})
    inputs = (Q, K, V, S, topk)
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    add_timing(res, t, 3)
    return res, inputs


def bench_prefill_interval(torch, hsa, args, inputs, R=8):
    """The 32K prefill workload with retrieval every R tokens (one selection
    per block of R tokens, per-token attention and fusion).  With R * G = 32
    the library runs it query-major: the invert and fusion stages are empty
    and the attend stage holds the fused attention."""
    Q, K, V, S, topk = inputs
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    q, k, v = to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch)
    out = torch.empty_like(q)
    ws = torch.empty(hsa.hsa_prefill_interval_workspace_size(B, L, Hq, Hkv, d, S, topk, R,
                                                             torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def step():
        hsa.hsa_prefill_interval(q, k, v, S, topk, R, out=out, workspace=ws)

    log(f"prefill, retrieval every {R} tokens: timing")
    t = time_steps(torch, hsa, step, args.steps, args.warmup, 5, args.flush)
    ms, stages = t["ms"], t["stage_mean"]
    n = L // S
    sel = sum(min(topk, min((t // R * R) // S, n)) for t in range(L))
    attn_flop = B * Hq * sel * S * d * 4
    attn_ms = stages[3]
    achieved = attn_flop / (attn_ms * 1e-3) / 1e12
    res = dict(
        value=B * L / (ms * 1e-3), unit="queries/s", ms_per_step=ms,
        config={"workload": f"hsa_prefill_r{R}", "B": B, "L": L, "Hq": Hq, "Hkv": Hkv, "d": d,
                "S": S, "topk": topk, "retrieval_interval": R,
                "inputs": "0.5*N(0,1) bf16, seed 2"},
        roofline={"bound": "mfma",
                  "kernel": "attend (query-major chunk attention with the fusion, bf16 MFMA; "
                            "the stage includes the landmark split)",
                  "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                  "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic_for("hsa_prefill_r8"),
                  "algorithmic_gflop_per_launch": attn_flop / 1e9, "avg_launch_ms": attn_ms,
                  "hbm_view": hbm_view(traffic_for("hsa_prefill_r8"), attn_ms)},
        stages_ms=dict(zip(["landmarks", "select", "invert", "attend", "fuse"], stages)))
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    add_timing(res, t, 3)
    return res


def bench_decode(torch, hsa, args, big=False):
    import numpy as np
    import synth
    if big:
        B, Hq, Hkv, N, d, S, topk, seed = 1, 16, 4, 16777216, 128, 64, 16, 4
    else:
        B, Hq, Hkv, N, d, S, topk, seed = 32, 32, 8, 131072, 128, 64, 8, 3
    log(f"decode: filling caches on the device (B={B}, N={N})")
    Kc = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device="cuda")
    Vc = torch.empty_like(Kc)
    synth.normal_device(Kc, seed, synth.TID_K)
    synth.normal_device(Vc, seed, synth.TID_V)
    qh = synth.normal((B, Hq, d), synth.BF16, seed, synth.TID_QDEC)
    if big:
        cstar = synth.pick_index(N // S, seed)
        G = Hq // Hkv
        for g in range(Hkv):
            key = synth.needle_key(qh[0, g * G:(g + 1) * G], True)
            rows = np.broadcast_to(key, (S, d)).copy()
            Kc[0, g, cstar * S:(cstar + 1) * S] = to_dev(rows, torch)
    q = to_dev(qh, torch)
    lmk = hsa.hsa_build_landmarks(Kc, S)
    out = torch.empty_like(q)
    ws = torch.empty(hsa.hsa_decode_workspace_size(B, Hq, Hkv, d, S, topk, N),
                     dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def step():
        hsa.hsa_decode(q, Kc, Vc, lmk, N, S, topk, out=out, workspace=ws)

    log("decode: timing")
    t = time_steps(torch, hsa, step, args.steps, args.warmup, 3, args.flush)
    ms, stages = t["ms"], t["stage_mean"]
    n = N // S
    lmk_bytes = B * Hkv * n * d * 4
    kv_bytes = B * Hkv * topk * S * d * 2 * 2
    qo_bytes = B * Hq * d * 2 * 2
    total = lmk_bytes + kv_bytes + qo_bytes
    scan_ms = stages[0]
    achieved = lmk_bytes / (scan_ms * 1e-3) / 1e9
    workload = "hsa_decode_16m" if big else "hsa_decode"
    res = dict(
        value=B / (ms * 1e-3), unit="queries/s", ms_per_step=ms,
        config={"workload": workload, "B": B, "n_ctx": N,
                "Hq": Hq, "Hkv": Hkv, "d": d, "S": S, "topk": topk,
                "inputs": f"N(0,1) bf16, seed {seed}" + (", planted needle" if big else "")},
        roofline={"bound": "hbm", "kernel": "scan (landmark stream + top-K)",
                  "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                  "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic_for(workload),
                  "algorithmic_bytes_per_launch": lmk_bytes, "avg_launch_ms": scan_ms},
        stages_ms=dict(zip(["scan", "attend", "fuse"], stages)),
        whole_path={"algorithmic_bytes": total, "gbps": total / (ms * 1e-3) / 1e9,
                    "hbm_frac": total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS})
    del Kc, Vc, lmk, q, out, ws
    torch.cuda.empty_cache()
    add_timing(res, t, 0)
    return res


def bench_dhsa(torch, hsa, args):
    import synth
    B, H, L, d, budget, seed = 1, 8, 16384, 128, 2048, 5
    offs = synth.chunk_offsets(L, 16, 128, seed=seed)
    Q = synth.normal((B, H, L, d), synth.BF16, seed, synth.TID_Q)
    K = synth.normal((B, H, L, d), synth.BF16, seed, synth.TID_K)
    V = synth.normal((B, H, L, d), synth.BF16, seed, synth.TID_V)
    q, k, v = to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch)
    out = torch.empty_like(q)
    ws = torch.empty(hsa.dhsa_prefill_workspace_size(B, L, H, d, len(offs) - 1, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def step():
        hsa.dhsa_prefill(q, k, v, offs, budget, out=out, workspace=ws)

    log("dhsa: timing")
    t = time_steps(torch, hsa, step, args.steps, args.warmup, 4, args.flush)
    ms, stages = t["ms"], t["stage_mean"]
    pairs = sum(min(budget, i + 1) for i in range(L))
    attn_flop = B * H * pairs * d * 4
    achieved = attn_flop / (stages[2] * 1e-3) / 1e12
    res = dict(
        value=B * L / (ms * 1e-3), unit="queries/s", ms_per_step=ms,
        config={"workload": "dhsa_prefill", "B": B, "L": L, "H": H, "d": d, "budget": budget,
                "chunks": len(offs) - 1, "inputs": "N(0,1) bf16, lengths U{16..128}, seed 5"},
        roofline={"bound": "mfma", "kernel": "attend (block-sparse masked attention)",
                  "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                  "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic_for("dhsa_prefill"),
                  "algorithmic_gflop_per_launch": attn_flop / 1e9, "avg_launch_ms": stages[2],
                  "hbm_view": hbm_view(traffic_for("dhsa_prefill"), stages[2])},
        stages_ms=dict(zip(["pool", "rank", "attend", "mask"], stages)))
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    add_timing(res, t, 2)
    return res


def bench_dhsa_decode(torch, hsa, args):
    """The 16K-token DHSA sequence decoding its last token (its last chunk is
    the current one), batch 32, 8 heads, N_b = 2048."""
    import synth
    B, H, L, d, budget, seed = 32, 8, 16384, 128, 2048, 5
    offs_all = synth.chunk_offsets(L, 16, 128, seed=seed)
    offs = offs_all[:-1]
    n = len(offs) - 1
    m = int(offs_all[-1] - offs_all[-2])
    log(f"dhsa decode: filling caches on the device (B={B}, L={L})")
    Kc = torch.empty((B, H, L, d), dtype=torch.bfloat16, device="cuda")
    Vc = torch.empty_like(Kc)
    synth.normal_device(Kc, seed, synth.TID_K)
    synth.normal_device(Vc, seed, synth.TID_V)
    qcur = to_dev(synth.normal((B, H, m, d), synth.BF16, seed, synth.TID_QDEC), torch)
    khat = hsa.dhsa_build_chunk_keys(Kc, offs)
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(hsa.dhsa_decode_workspace_size(B, H, d, n, budget, L), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()

    def step():
        hsa.dhsa_decode(qcur, Kc, Vc, khat, offs, budget, out=out, workspace=ws)

    log("dhsa decode: timing")
    t = time_steps(torch, hsa, step, args.steps, args.warmup, 3, args.flush)
    ms, stages = t["ms"], t["stage_mean"]
    pos = L - 1
    kept = min(budget, pos + 1)
    kv_bytes = B * H * kept * d * 2 * 2            # the kept keys and values
    khat_bytes = B * H * n * d * 4                 # pooled keys of the complete chunks
    cur_bytes = B * H * m * d * 2 * 2              # current chunk's queries and keys
    total = kv_bytes + khat_bytes + cur_bytes + B * H * d * 2
    achieved = kv_bytes / (stages[1] * 1e-3) / 1e9
    res = dict(
        value=B / (ms * 1e-3), unit="queries/s", ms_per_step=ms,
        config={"workload": "dhsa_decode", "B": B, "H": H, "d": d, "context": L,
                "complete_chunks": n, "current_chunk": m, "budget": budget,
                "inputs": "N(0,1) bf16, lengths U{16..128}, seed 5"},
        roofline={"bound": "hbm", "kernel": "attend (gather of the kept keys and values)",
                  "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                  "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic_for("dhsa_decode"),
                  "algorithmic_bytes_per_launch": kv_bytes, "avg_launch_ms": stages[1]},
        stages_ms=dict(zip(["score", "attend", "combine"], stages)),
        whole_path={"algorithmic_bytes": total, "gbps": total / (ms * 1e-3) / 1e9,
                    "hbm_frac": total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS})
    del Kc, Vc, qcur, khat, out, ws
    torch.cuda.empty_cache()
    add_timing(res, t, 1)
    return res


def bench_backward(torch, hsa, args, inputs):
    """HSA prefill backward on the 32K prefill workload: gradients of
    sum(dO * O) for an N(0,1) bf16 output gradient."""
    import synth
    Q, K, V, S, topk = inputs
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    q, k, v = to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch)
    dO = to_dev(synth.normal((B, Hq, L, d), synth.BF16, 2, synth.TID_DO), torch)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = torch.empty(hsa.hsa_prefill_backward_workspace_size(B, L, Hq, Hkv, d, S, topk,
                                                             torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def step():
        hsa.hsa_prefill_backward(q, k, v, dO, S, topk, workspace=ws, grads=grads)

    log("backward: timing")
    t = time_steps(torch, hsa, step, args.steps, args.warmup, 8, args.flush)
    ms, stages = t["ms"], t["stage_mean"]
    sel, _ = prefill_counts(L, S, topk)
    rows = B * Hq * sel  # (token, head, selected chunk) rows
    # kv stage per row: S = Q K^T, dP = dO V^T, dV and dK products
    kv_flop = rows * S * d * 2 * 4
    achieved = kv_flop / (stages[6] * 1e-3) / 1e12
    res = dict(
        value=B * L / (ms * 1e-3), unit="queries/s", ms_per_step=ms,
        config={"workload": "hsa_prefill_backward", "B": B, "L": L, "Hq": Hq, "Hkv": Hkv,
                "d": d, "S": S, "topk": topk, "inputs": "0.5*N(0,1) bf16 Q/K/V, N(0,1) dO, seed 2"},
        roofline={"bound": "mfma", "kernel": "kv (dK, dV; bf16 MFMA)",
                  "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                  "frac": achieved / PEAK_BF16_TFLOPS,
                  "traffic": traffic_for("hsa_prefill_backward"),
                  "algorithmic_gflop_per_launch": kv_flop / 1e9, "avg_launch_ms": stages[6],
                  "hbm_view": hbm_view(traffic_for("hsa_prefill_backward"), stages[6])},
        stages_ms=dict(zip(["landmarks", "select", "invert", "weights", "score", "rows", "kv",
                            "finish"], stages)))
    del q, k, v, dO, grads, ws
    torch.cuda.empty_cache()
    add_timing(res, t, 6)
    return res


def bench_swa(torch, hsa, args, inputs, W=512):
    """Sliding-window attention of the upper layers over the 32K prefill
    workload's Q, K, V (512-token window)."""
    Q, K, V, _, _ = inputs
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    q, k, v = to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch)
    out = torch.empty_like(q)

    def step():
        hsa.swa_prefill(q, k, v, W, out=out)

    log(f"swa prefill (W={W}): timing")
    t = time_steps(torch, hsa, step, args.steps, args.warmup, 1, args.flush)
    ms, stages = t["ms"], t["stage_mean"]
    pairs = sum(min(W, t + 1) for t in range(L))
    flop = B * Hq * pairs * d * 4
    achieved = flop / (stages[0] * 1e-3) / 1e12
    res = dict(
        value=B * L / (ms * 1e-3), unit="queries/s", ms_per_step=ms,
        config={"workload": "swa_prefill", "B": B, "L": L, "Hq": Hq, "Hkv": Hkv, "d": d,
                "window": W, "inputs": "0.5*N(0,1) bf16, seed 2"},
        roofline={"bound": "mfma", "kernel": "sliding-window attention (bf16 MFMA)",
                  "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                  "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic_for("swa_prefill"),
                  "algorithmic_gflop_per_launch": flop / 1e9, "avg_launch_ms": stages[0],
                  "hbm_view": hbm_view(traffic_for("swa_prefill"), stages[0])},
        stages_ms={"attend": stages[0]})
    del q, k, v, out
    torch.cuda.empty_cache()
    add_timing(res, t, 0)
    return res


def bench_swa_decode(torch, hsa, args, W=512):
    """Sliding-window decode at the end of 131072-token caches, batch 32,
    32 query heads over 8 KV heads (the HSA decode workload's shapes)."""
    import synth
    B, Hq, Hkv, N, d, seed = 32, 32, 8, 131072, 128, 3
    log(f"swa decode: filling caches on the device (B={B}, N={N})")
    Kc = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device="cuda")
    Vc = torch.empty_like(Kc)
    synth.normal_device(Kc, seed, synth.TID_K)
    synth.normal_device(Vc, seed, synth.TID_V)
    q = to_dev(synth.normal((B, Hq, d), synth.BF16, seed, synth.TID_QDEC), torch)
    out = torch.empty_like(q)
    torch.cuda.synchronize()

    def step():
        hsa.swa_decode(q, Kc, Vc, N - 1, W, out=out)

    log("swa decode: timing")
    t = time_steps(torch, hsa, step, args.steps, args.warmup, 1, args.flush)
    ms, stages = t["ms"], t["stage_mean"]
    kv_bytes = B * Hkv * W * d * 2 * 2
    total = kv_bytes + B * Hq * d * 2 * 2
    achieved = total / (stages[0] * 1e-3) / 1e9
    res = dict(
        value=B / (ms * 1e-3), unit="queries/s", ms_per_step=ms,
        config={"workload": "swa_decode", "B": B, "n_ctx": N, "Hq": Hq, "Hkv": Hkv, "d": d,
                "window": W, "inputs": f"N(0,1) bf16, seed {seed}"},
        roofline={"bound": "hbm", "kernel": "sliding-window decode (window keys and values)",
                  "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                  "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic_for("swa_decode"),
                  "algorithmic_bytes_per_launch": total, "avg_launch_ms": stages[0]},
        stages_ms={"attend": stages[0]})
    del Kc, Vc, q, out
    torch.cuda.empty_cache()
    add_timing(res, t, 0)
    return res


def bench_upper_prefill(torch, hsa, args, inputs, W=512):
    """The upper layers' two attentions over the 32K prefill workload in one
    pass (hsa_swa_prefill): HSA prefill and 512-token sliding-window
    attention of the same Q, K, V, their attention blocks in one launch.  The
    same two outputs from separate hsa_prefill and swa_prefill calls are
    timed beside it."""
    Q, K, V, S, topk = inputs
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    q, k, v = to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch)
    oh, osw = torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(hsa.hsa_prefill_workspace_size(B, L, Hq, Hkv, d, S, topk, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def step():
        hsa.hsa_swa_prefill(q, k, v, S, topk, W, out_hsa=oh, out_swa=osw, workspace=ws)

    def separate():
        hsa.hsa_prefill(q, k, v, S, topk, out=oh, workspace=ws)
        hsa.swa_prefill(q, k, v, W, out=osw)

    log(f"upper-layer prefill (W={W}): timing")
    t = time_steps(torch, hsa, step, args.steps, args.warmup, 5, args.flush)
    ms, stages = t["ms"], t["stage_mean"]
    t_sep = time_steps(torch, hsa, separate, args.steps, args.warmup, 6, args.flush)
    sel, _ = prefill_counts(L, S, topk)
    hsa_flop = B * Hq * sel * S * d * 4
    swa_flop = B * Hq * sum(min(W, t_ + 1) for t_ in range(L)) * d * 4
    flop = hsa_flop + swa_flop
    achieved = flop / (stages[3] * 1e-3) / 1e12
    res = dict(
        value=B * L / (ms * 1e-3), unit="queries/s", ms_per_step=ms,
        config={"workload": "hsa_swa_prefill", "B": B, "L": L, "Hq": Hq, "Hkv": Hkv, "d": d,
                "S": S, "topk": topk, "window": W, "inputs": "0.5*N(0,1) bf16, seed 2"},
        roofline={"bound": "mfma", "kernel": "attend (HSA chunk attention and sliding-window "
                                             "attention in one launch, bf16 MFMA)",
                  "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                  "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                  "algorithmic_gflop_per_launch": flop / 1e9, "avg_launch_ms": stages[3]},
        stages_ms=dict(zip(["landmarks", "select", "invert", "attend", "fuse"], stages)),
        separate_calls_ms=t_sep["ms"])
    add_timing(res, t, 3)
    del q, k, v, oh, osw, ws
    torch.cuda.empty_cache()
    return res


def bench_upper_decode(torch, hsa, args, W=512):
    """The upper layers' two attentions of one new query in one pass
    (hsa_swa_decode): HSA decode and 512-token sliding-window decode at the
    end of 131072-token caches, batch 32, 32 query heads over 8 KV heads,
    S = 64, top-8.  The same two outputs from separate hsa_decode and
    swa_decode calls are timed beside it."""
    import synth
    B, Hq, Hkv, N, d, S, topk, seed = 32, 32, 8, 131072, 128, 64, 8, 3
    n_ctx = N - 1  # the new token's key and value are the cache's last row
    log(f"upper-layer decode: filling caches on the device (B={B}, N={N})")
    Kc = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device="cuda")
    Vc = torch.empty_like(Kc)
    synth.normal_device(Kc, seed, synth.TID_K)
    synth.normal_device(Vc, seed, synth.TID_V)
    q = to_dev(synth.normal((B, Hq, d), synth.BF16, seed, synth.TID_QDEC), torch)
    lmk = hsa.hsa_build_landmarks(Kc, S)
    oh, osw = torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(hsa.hsa_swa_decode_workspace_size(B, Hq, Hkv, d, S, topk, n_ctx, W),
                     dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def step():
        hsa.hsa_swa_decode(q, Kc, Vc, lmk, n_ctx, S, topk, W, out_hsa=oh, out_swa=osw,
                           workspace=ws)

    def separate():
        hsa.hsa_decode(q, Kc, Vc, lmk, n_ctx, S, topk, out=oh, workspace=ws)
        hsa.swa_decode(q, Kc, Vc, n_ctx, W, out=osw)

    log(f"upper-layer decode (W={W}): timing")
    t = time_steps(torch, hsa, step, args.steps, args.warmup, 3, args.flush)
    ms, stages = t["ms"], t["stage_mean"]
    t_sep = time_steps(torch, hsa, separate, args.steps, args.warmup, 4, args.flush)
    n = n_ctx // S
    lmk_bytes = B * Hkv * n * d * 4
    kv_bytes = B * Hkv * topk * S * d * 2 * 2
    win_bytes = B * Hkv * W * d * 2 * 2
    qo_bytes = B * Hq * d * 2 * 3
    total = lmk_bytes + kv_bytes + win_bytes + qo_bytes
    res = dict(
        value=B / (ms * 1e-3), unit="queries/s", ms_per_step=ms,
        config={"workload": "hsa_swa_decode", "B": B, "n_ctx": n_ctx, "Hq": Hq, "Hkv": Hkv,
                "d": d, "S": S, "topk": topk, "window": W, "inputs": f"N(0,1) bf16, seed {seed}"},
        roofline={"bound": "hbm", "kernel": "whole step (landmark stream, chunk and window "
                                            "gathers)",
                  "achieved": total / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                  "frac": total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, "traffic": None,
                  "algorithmic_bytes_per_launch": total, "avg_launch_ms": ms},
        stages_ms=dict(zip(["scan", "attend", "fuse"], stages)),
        separate_calls_ms=t_sep["ms"])
    res["ms_per_step_mean"] = t["ms_mean"]
    del Kc, Vc, q, lmk, oh, osw, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(inputs, target_s):
    """The oracle as it is, timed on this host's cores on evenly spaced query
    positions of the prefill workload (every head), scaled to queries/s."""
    import numpy as np
    import oracle
    Q, K, V, S, topk = inputs
    L = Q.shape[2]
    probe = np.arange(0, L, L // 64)
    t0 = time.perf_counter()
    oracle.hsa_prefill(Q, K, V, S, topk, rows=probe)
    per_row = (time.perf_counter() - t0) / len(probe)
    n_rows = int(min(L, max(64, target_s / max(per_row, 1e-9))))
    rows = np.linspace(0, L - 1, n_rows).astype(np.int64)
    log(f"cpu baseline: {n_rows} rows on {oracle.num_threads()} threads")
    t0 = time.perf_counter()
    oracle.hsa_prefill(Q, K, V, S, topk, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": n_rows / dt, "unit": "queries/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": dt,
            "sample": f"{n_rows} of {L} query positions, evenly spaced, all 16 heads, "
                      "double precision C oracle (OpenMP)"}


def _counter_rows(run_dir):
    """(dispatch id, kernel name, value) of a rocprofv3 --pmc csv run."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"{run_dir}: expected one *counter_collection.csv, found {len(files)}")
    rows = []
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return rows


def summarize_counters(fetch_dir, write_dir, bench_json):
    """Per-launch HBM bytes of each workload's dominant kernel from a
    FETCH_SIZE run and a WRITE_SIZE run (KiB per dispatch) of the same bench
    command, each scaled by what the counter reads for the trailing plain
    copy of known size (--copy-calibration)."""
    with open(bench_json) as fh:
        line = json.loads(fh.read().strip().splitlines()[-1])
    order = [line["config"]["workload"]] + [a["config"]["workload"]
                                           for a in line.get("also", [])]
    per = line["warmup"] + 2 * line["steps"]  # warm-up, timed and per-stage passes
    cal = line.get("copy_calibration_bytes")
    if not cal:
        raise SystemExit("the bench run needs --copy-calibration")
    out = {"calibration_copy_bytes": cal, "launches_per_workload": per, "workloads": {}}
    vals = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d)
        copies = [v for _, n, v in rows if "copy" in n.lower()][-2:]
        scale = cal / (sum(copies) / len(copies) * 1024.0)
        out[counter.lower() + "_scale"] = scale
        used = {}
        for w in order:
            if w not in DOMINANT:
                continue
            name, args_t = DOMINANT[w][0], DOMINANT[w][1]
            mine = [v for _, n, v in rows if name in n and args_t in n]
            k0 = used.get((name, args_t), 0)
            take = mine[k0:k0 + per]
            used[(name, args_t)] = k0 + per
            if len(take) != per:
                raise SystemExit(f"{counter}: {w}: expected {per} launches of {name}")
            vals.setdefault(w, {})[counter] = sum(take) / per
    for w, v in vals.items():
        f_b = v["FETCH_SIZE"] * 1024.0 * out["fetch_size_scale"]
        w_b = v["WRITE_SIZE"] * 1024.0 * out["write_size_scale"]
        out["workloads"][w] = {"kernel": DOMINANT[w][0], "fetch_kib_per_launch": v["FETCH_SIZE"],
                               "write_kib_per_launch": v["WRITE_SIZE"], "fetch_bytes": f_b,
                               "write_bytes": w_b, "traffic_bytes": f_b + w_b,
                               "sources_sha1": sources_sha1(w)}
    # secondary kernels: each launches once per call of its workload too
    out["secondary"] = {}
    for w, (name, args_t, _) in SECONDARY.items():
        if w not in order:
            continue
        rec = {"kernel": name, "sources_sha1": sources_sha1(w, SECONDARY)}
        for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
            rows = _counter_rows(d)
            mine = [val for _, n, val in rows if name in n and args_t in n]
            k0 = sum(per for x in order[:order.index(w)]
                     if x in SECONDARY and SECONDARY[x][:2] == (name, args_t))
            take = mine[k0:k0 + per]
            if len(take) != per:
                raise SystemExit(f"{counter}: {w}: expected {per} launches of {name}")
            scale = out[counter.lower() + "_scale"]
            rec[counter.lower() + "_bytes"] = sum(take) / per * 1024.0 * scale
        rec["traffic_bytes"] = rec["fetch_size_bytes"] + rec["write_size_bytes"]
        out["secondary"][w] = rec
    return out


def _trace_rows(run_dir):
    """(start ns, end ns, kernel name) of every dispatch of a rocprofv3
    --kernel-trace csv run, in dispatch order."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"{run_dir}: expected one *kernel_trace.csv, found {len(files)}")
    rows = []
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            rows.append((int(r["Dispatch_Id"]), int(r["Start_Timestamp"]),
                         int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    return [(a, b, n) for _, a, b, n in rows]


def summarize_trace(trace_dir, bench_json):
    """Per-workload launch durations of each dominant kernel from a rocprofv3
    --kernel-trace run of one bench command, beside the HIP-event average the
    same run reported: workloads run in order and each launches its dominant
    kernel warmup + 2 * steps times (warm-up, timed and per-stage passes), so
    the trace's launches are attributed in that order.  The last `steps`
    launches of each workload are the per-stage pass the events timed."""
    with open(bench_json) as fh:
        line = json.loads(fh.read().strip().splitlines()[-1])
    recs = [line] + line.get("also", [])
    per = line["warmup"] + 2 * line["steps"]
    rows = _trace_rows(trace_dir)
    used, out = {}, []
    for rec in recs:
        w = rec["config"]["workload"]
        if w not in DOMINANT:
            continue
        name, args_t = DOMINANT[w][0], DOMINANT[w][1]
        mine = [(b - a) / 1e3 for a, b, n in rows if name in n and args_t in n]
        k0 = used.get((name, args_t), 0)
        take = mine[k0:k0 + per]
        used[(name, args_t)] = k0 + per
        if len(take) != per:
            raise SystemExit(f"{w}: expected {per} launches of {name}, found {len(take)}")
        staged = take[-line["steps"]:]
        ev_us = rec["roofline"]["avg_launch_ms"] * 1e3
        out.append({"workload": w, "kernel": name, "launches": per,
                    "trace_avg_us_all": sum(take) / per,
                    "trace_avg_us_stage_pass": sum(staged) / len(staged),
                    "trace_median_us_stage_pass": _median(staged),
                    "event_avg_us": ev_us,
                    "event_vs_trace": ev_us / (sum(staged) / len(staged))})
    return out


def summarize_sq(run_dir, bench_json):
    """Per-workload SQ counters of each dominant kernel from a rocprofv3 --pmc
    run (MfmaUtil, VALUBusy, SQ_INSTS_VALU_MFMA_MOPS_BF16) of one bench
    command: MFMA-busy and VALU-busy percentages averaged over the workload's
    launches, and the bf16 MFMA flops the kernel executed (MOPS * 512)
    against the algorithmic flops of the record."""
    import csv
    import glob
    with open(bench_json) as fh:
        line = json.loads(fh.read().strip().splitlines()[-1])
    recs = [line] + line.get("also", [])
    per = line["warmup"] + 2 * line["steps"]
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"{run_dir}: expected one *counter_collection.csv, found {len(files)}")
    by_disp = {}
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            d = by_disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    disp = [by_disp[k] for k in sorted(by_disp)]
    used, out = {}, []
    for rec in recs:
        w = rec["config"]["workload"]
        if w not in DOMINANT or rec["roofline"]["bound"] != "mfma":
            continue
        name, args_t = DOMINANT[w][0], DOMINANT[w][1]
        mine = [d for d in disp if name in d["name"] and args_t in d["name"]]
        k0 = used.get((name, args_t), 0)
        take = mine[k0:k0 + per]
        used[(name, args_t)] = k0 + per
        if len(take) != per:
            raise SystemExit(f"{w}: expected {per} launches of {name}, found {len(take)}")
        avg = {c: sum(d.get(c, 0.0) for d in take) / per
               for c in ("MfmaUtil", "VALUBusy", "SQ_INSTS_VALU_MFMA_MOPS_BF16")}
        alg = rec["roofline"]["algorithmic_gflop_per_launch"] * 1e9
        executed = avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        out.append({"workload": w, "kernel": name, "launches": per,
                    "mfma_busy_pct": avg["MfmaUtil"], "valu_busy_pct": avg["VALUBusy"],
                    "executed_mfma_gflop": executed / 1e9, "algorithmic_gflop": alg / 1e9,
                    "executed_over_algorithmic": executed / alg if alg else None,
                    "algorithmic_mfma_frac": rec["roofline"]["frac"],
                    "sources_sha1": sources_sha1(w)})
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--extras", default="prefill_r8,backward,decode,decode16m,dhsa,dhsa_decode,"
                                        "swa,swa_decode,upper_prefill,upper_decode",
                    help="comma list of extra workloads: prefill_r8, backward, decode, "
                         "decode16m, dhsa, dhsa_decode, swa, swa_decode, upper_prefill, "
                         "upper_decode, or none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-mode", choices=["write-read", "write"], default="write-read",
                    help="cache flush before each timed call: a 1 GiB write, then a read of it "
                         "(default), or the write alone")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="after the workloads, copy GIB GiB device-to-device twice (a plain "
                         "copy kernel of known size to scale HBM byte counters)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_RUN_DIR", "BENCH_JSON"),
                    help="no GPU work: per-workload launch durations of the dominant kernels "
                         "from a rocprofv3 --kernel-trace run of one bench command")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("PMC_RUN_DIR", "BENCH_JSON"),
                    help="no GPU work: per-workload MFMA/VALU busy and executed MFMA flops of "
                         "the dominant kernels from a rocprofv3 --pmc MfmaUtil VALUBusy "
                         "SQ_INSTS_VALU_MFMA_MOPS_BF16 run of one bench command")
    ap.add_argument("--summarize-counters", nargs=3,
                    metavar=("FETCH_RUN_DIR", "WRITE_RUN_DIR", "BENCH_JSON"),
                    help="no GPU work: summarise two rocprofv3 --pmc runs (FETCH_SIZE, "
                         "WRITE_SIZE) of one bench command with --copy-calibration, and print "
                         "per-launch HBM traffic of each workload's dominant kernel")
    args = ap.parse_args()
    if args.summarize_counters:
        print(json.dumps(summarize_counters(*args.summarize_counters), indent=1))
        return
    if args.summarize_trace:
        print(json.dumps(summarize_trace(*args.summarize_trace), indent=1))
        return
    if args.summarize_sq:
        print(json.dumps(summarize_sq(*args.summarize_sq), indent=1))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(see the sharding notes in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunk_hierarchical_sparse_amd as hsa

    torch.cuda.set_device(0)
    args.flush = Flush(torch, mode=args.flush_mode)
    args.copy_rate = measure_copy_rate(torch, args.flush)
    res, inputs = bench_prefill(torch, hsa, args)
    line = {"metric": METRIC, "value": res["value"], "unit": "queries/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic", "config": res["config"], "roofline": res["roofline"],
            "stages_ms": res["stages_ms"], "whole_path": res["whole_path"],
            "traffic_floor": res["traffic_floor"],
            "ms_per_step_mean": res["ms_per_step_mean"],
            "timing": "median of K steps, each between its own HIP events on the library's "
                      "stream after " + args.flush.describe() + ", outside the events"}
    also = []
    extras = [e for e in args.extras.split(",") if e and e != "none"]
    for e in extras:
        if e == "prefill_r8":
            also.append(bench_prefill_interval(torch, hsa, args, inputs))
        elif e == "decode":
            also.append(bench_decode(torch, hsa, args))
        elif e == "decode16m":
            also.append(bench_decode(torch, hsa, args, big=True))
        elif e == "dhsa":
            also.append(bench_dhsa(torch, hsa, args))
        elif e == "dhsa_decode":
            also.append(bench_dhsa_decode(torch, hsa, args))
        elif e == "backward":
            also.append(bench_backward(torch, hsa, args, inputs))
        elif e == "swa":
            also.append(bench_swa(torch, hsa, args, inputs))
        elif e == "swa_decode":
            also.append(bench_swa_decode(torch, hsa, args))
        elif e == "upper_prefill":
            also.append(bench_upper_prefill(torch, hsa, args, inputs))
        elif e == "upper_decode":
            also.append(bench_upper_decode(torch, hsa, args))
        else:
            raise SystemExit(f"unknown extra workload {e}")
    if also:
        line["also"] = also
    if args.copy_calibration > 0:
        n = int(args.copy_calibration * (1 << 30))
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inputs, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
