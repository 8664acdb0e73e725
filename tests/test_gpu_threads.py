"""GPU: the library's first launches from several host threads at once.

Each scan kernel is prepared once per device before its first launch (the scratch check and the raised
dynamic-LDS cap, under a lock).  A fresh process starts four threads that call ssd_chunk_scan_fwd together
(bf16 with the split workspace: the pre-pass and the full pass; fp32 without a workspace), each on its own
inputs' copy and outputs; every call must succeed and equal, bit for bit, the same call made afterwards from
the main thread.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys, threading
sys.path.insert(0, sys.argv[1])
import torch
import selective_state_space_14_amd as ssd
import synth

dev = "cuda"
cases = [synth.Workload("thr_bf16", 2, 1000, 8, 64, 64, 2, "bf16", conv=False),
         synth.Workload("thr_f32", 2, 300, 4, 64, 32, 1, "f32", conv=False)]

def setup(wl, seed):
    prm = synth.params(wl, seed, device=dev)
    ins = synth.scan_inputs(wl, seed, device=dev)
    code = ssd.SSD_BF16 if wl.dtype == "bf16" else ssd.SSD_F32
    nb = ssd.ssd_chunk_scan_workspace_size(wl.B, wl.L, wl.H, wl.P, wl.N, wl.G, code) if wl.dtype == "bf16" else 0
    ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    return prm, ins, ws, nb

def run(wl, prm, ins, ws):
    fs = torch.empty(wl.B, wl.H, wl.P, wl.N, device=dev)
    y = ssd.ssd_chunk_scan_fwd(ins["x"], ins["Bm"], ins["Cm"], ins["dt_raw"], prm["A"], H=wl.H, P=wl.P, N=wl.N,
                               G=wl.G, D=prm["D"], z=ins["z"], final_state=fs, workspace=ws, dt_softplus=True,
                               dt_bias=prm["dt_bias"])
    return y, fs

jobs = []
for wl in cases:
    for k in range(2):
        jobs.append((wl,) + setup(wl, 3))
torch.cuda.synchronize()
assert any(nb > 0 for _, _, _, _, nb in jobs), "the bf16 case must take the split path"
out = [None] * len(jobs)
err = []
gate = threading.Barrier(len(jobs))

def work(i):
    wl, prm, ins, ws, _ = jobs[i]
    try:
        gate.wait()
        out[i] = run(wl, prm, ins, ws)
    except Exception as e:
        err.append(repr(e))

ts = [threading.Thread(target=work, args=(i,)) for i in range(len(jobs))]
for t in ts: t.start()
for t in ts: t.join()
torch.cuda.synchronize()
assert not err, err
for i, (wl, prm, ins, ws, _) in enumerate(jobs):
    y, fs = run(wl, prm, ins, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, out[i][0]) and torch.equal(fs, out[i][1]), (wl.name, i)
print("threads ok", len(jobs), flush=True)
'''


def test_first_launches_from_several_threads():
    print("first launches from four host threads (fresh process)", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "threads ok 4" in r.stdout
