"""The timeline build (measurement tool) on the GPU: a small Gram NS call
through libgns_timeline.so, in a child process (one process cannot load both
library builds).  Every GEMM launch of the call leaves exactly one record per
workgroup of its grid, each workgroup's four stamps are in order, and the
call's output equals the library build's bit for bit (the timestamps change
no arithmetic)."""
import os
import subprocess
import sys

import pytest
import torch

from gpu_common import NS5, need_gpu, say
from gram_newton_schulz_amd import build, synth

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import sys, json
import numpy as np, torch
sys.path.insert(0, sys.argv[1])
from gram_newton_schulz_amd import timeline, binding, synth
L = timeline.timeline_lib()
X = torch.load(sys.argv[2], weights_only=True).cuda()
binding.timing_reset(); binding.timing_enable(True)
timeline.reset_records(L)
out = binding.gram_ns_batched(X, synth.NS5_MUON, (2,), split_batch=False)
torch.cuda.synchronize()
r = timeline.read_records(L)
launch_names = [rec[1] for rec in binding.timing_read() if rec[1].startswith("gemm")]
torch.save(out.cpu(), sys.argv[3])
f = timeline._fields(r)
groups = timeline.launches(f)
print(json.dumps({
    "records": int(len(r)),
    "gemm_launches": len(launch_names),
    "groups": [int(len(g)) for g in groups],
    "grids": [int(f["grid"][g[0]]) for g in groups],
    "ordered": bool(np.all(f["t0"] <= f["t1"]) and np.all(f["t1"] <= f["t2"]) and np.all(f["t2"] <= f["t3"])),
}))
"""


def test_timeline_records_every_workgroup(tmp_path):
    gns = need_gpu()
    if not os.path.exists(build.TIMELINE_LIB):
        pytest.skip("timeline build not present (python -m gram_newton_schulz_amd.build --timeline)")
    X = synth.batch(4, 512, 1536, seed=91, dtype=torch.bfloat16)       # 256-edge tiles, one stream
    xin, xout = tmp_path / "x.pt", tmp_path / "out.pt"
    torch.save(X, xin)
    say("timeline child process")
    res = subprocess.run([sys.executable, "-c", _CHILD, ROOT, str(xin), str(xout)], capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    import json
    d = json.loads(res.stdout.strip().splitlines()[-1])
    say("  ", d)
    assert d["ordered"]
    assert d["records"] == sum(d["groups"])
    assert len(d["groups"]) == d["gemm_launches"]
    assert d["groups"] == d["grids"]                   # one record per workgroup of every launch
    ref = gns.gram_ns_batched(X.cuda(), NS5, restarts=(2,), split_batch=False)
    torch.cuda.synchronize()
    assert torch.equal(torch.load(xout, weights_only=True), ref.cpu())
