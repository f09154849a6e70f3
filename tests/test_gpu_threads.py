"""Host threads: the first launches of every kernel family race from eight
threads at once (each on its own stream) in a fresh process, where the
launchers fill their per-device occupancy caches; every output must equal a
sequential rerun bit for bit (the kernels are deterministic)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, threading
sys.path.insert(0, sys.argv[1])
import torch
import causal_attention_score_amd as cas
from causal_attention_score_amd import synth

NT = 8
torch.manual_seed(0)
jobs = []
for i in range(NT):
    dt = (torch.float32, torch.bfloat16)[i % 2]
    B, T, NH, HS = 2, 300 + 129 * i, 3, 64
    qkv = torch.randn(B, T, 3 * NH * HS, device="cuda").to(dt)
    x = torch.randn(200 + 17 * i, 136, device="cuda").to(dt)
    w = torch.randn(150 + 5 * i, 136, device="cuda").to(dt)
    jobs.append((qkv, NH, x, w))
torch.cuda.synchronize()

def run(job):
    # scores, the fused softmax, the two-launch softmax (statistics, rows), the dense product
    qkv, NH, x, w = job
    outs = [cas.trimul_causal(qkv, NH)]
    outs += list(cas.causal_softmax(qkv, NH, fused=True))
    outs += list(cas.causal_softmax(qkv, NH, fused=False))
    outs.append(cas.gemm_nt(x, w))
    return outs

streams = [torch.cuda.Stream() for _ in range(NT)]
results = [None] * NT
gate = threading.Barrier(NT)

def work(i):
    gate.wait()
    with torch.cuda.stream(streams[i]):
        results[i] = run(jobs[i])
    streams[i].synchronize()

threads = [threading.Thread(target=work, args=(i,)) for i in range(NT)]
for t in threads:
    t.start()
for t in threads:
    t.join()
torch.cuda.synchronize()
bad = 0
for i in range(NT):
    again = run(jobs[i])
    torch.cuda.synchronize()
    for a, b in zip(results[i], again):
        if not torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)):
            bad += 1
print("threads ok" if bad == 0 else f"threads mismatch {bad}", flush=True)
sys.exit(1 if bad else 0)
"""


def test_concurrent_first_launches():
    print("case: eight host threads, first launches", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "threads ok" in r.stdout
