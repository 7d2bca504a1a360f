"""HSA_ATTN_LOG on the GPU: a child process with the variable set runs one
small hsa_prefill and hsa_decode; stderr must carry the entry-point line
and one launch line per kernel, with the instantiated kernel names."""
import os
import re
import subprocess
import sys

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import torch
import chunk_hierarchical_sparse_amd as hsa
g = torch.Generator(device="cuda").manual_seed(0)
Q = torch.randn(1, 8, 512, 128, device="cuda", generator=g).bfloat16()
K = torch.randn(1, 2, 512, 128, device="cuda", generator=g).bfloat16()
V = torch.randn(1, 2, 512, 128, device="cuda", generator=g).bfloat16()
out = hsa.hsa_prefill(Q, K, V, 64, 4)
lmk = hsa.hsa_build_landmarks(K, 64)
o = hsa.hsa_decode(Q[:, :, -1].contiguous(), K, V, lmk, 511, 64, 4)
torch.cuda.synchronize()
print("done", flush=True)
"""


def test_log_prints_entry_points_and_launches():
    say("HSA_ATTN_LOG child process")
    env = dict(os.environ, HSA_ATTN_LOG="1", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", SCRIPT], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "done" in r.stdout
    lines = [l for l in r.stderr.splitlines() if l.startswith("hsa_attn:")]
    text = "\n".join(lines)
    say(text)
    assert "hsa_attn: hsa_prefill B=1 L=512 Hq=8 Hkv=2 d=128 S=64 topk=4 dtype=1" in lines
    assert "hsa_attn: hsa_decode B=1 n_ctx=511 n_max=512 Hq=8 Hkv=2 d=128 S=64 topk=4 dtype=1" \
        in lines
    launch = re.compile(r"hsa_attn:   launch (\S.*) grid \((\d+), 1, 1\) block \((\d+), 1, 1\) "
                        r"lds (\d+) B$")
    names = [m.group(1) for m in map(launch.match, lines) if m]
    for want in ["select_mfma_kernel<128, 8>", "attend_chunk_bf16_kernel<128, true>",
                 "scan_kernel<128, 1>", "attend_fuse_kernel<128, 1>"]:
        assert want in names, (want, names)
    assert any(n.startswith("fuse_kernel<128, 1") for n in names), names
