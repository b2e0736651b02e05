"""Boundary promises that need a device: the hot calls allocate no device
memory (the one-time set-up is chol_init, or the first call), in a fresh
process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, sys.argv[1])
import torch
import differentiable_cholesky_amd as dc
import workloads

torch.cuda.init()


def free():
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


n = 1000
A = workloads.gram_spd(n, seed=3, device="cuda")
L = torch.empty_like(A)
info = torch.zeros(1, dtype=torch.int32, device="cuda")
adjL = torch.tril(torch.ones_like(A))
adjA = torch.zeros_like(A)
ws = torch.empty(dc.chol_potrf_adjoint_workspace_size(dc.CHOL_F64, n, 0, True, False), dtype=torch.uint8,
                 device="cuda")
Ab = (2.0 * torch.eye(32, device="cuda")).expand(64, 32, 32).contiguous()
Lb = torch.empty_like(Ab)
ib = torch.zeros(64, dtype=torch.int32, device="cuda")
Gb = torch.zeros_like(Ab)
f0 = free()
dc.chol_init()
f1 = free()
for _ in range(2):
    dc.chol_potrf(A, L, info)
    dc.chol_potrf_adjoint(L, adjL, adjA, accumulate=True, workspace=ws)
    dc.chol_potrf_batched(Ab, Lb, ib)
    dc.chol_potrf_adjoint_batched(Lb, Lb, Gb)
f2 = free()
print("init_bytes", f0 - f1, "call_bytes", f1 - f2, "info", int(info.item()), flush=True)
"""


def test_blocked_calls_allocate_no_device_memory_in_fresh_process():
    r = subprocess.run([sys.executable, "-c", SCRIPT, ROOT], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("init_bytes")][-1]
    f = line.split()
    print(line)
    assert int(f[5]) == 0
    assert int(f[3]) == 0, f"device memory changed across the calls: {line}"
