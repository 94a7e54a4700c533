"""OWQ_CHECK=1: the host re-checks weak_idx before packing or a linear and
reports OWQ_ERR_RANGE for indices that are not strictly ascending in [0, K).
The variable is read once per process, so the check runs in a child process;
the error is found on the host, before anything is enqueued."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import torch
from mixed_precision_weight_amd import owq
W = (0.02 * torch.randn(64, 96)).half().cuda()
x = torch.randn(1, 96).half().cuda()
good = torch.tensor([3, 40], dtype=torch.int32, device="cuda")
p = owq.pack(W, good)
owq.linear(p, x)
print("GOOD OK", flush=True)
for bad in ([40, 3], [3, 3], [3, 96], [-1, 3]):
    idx = torch.tensor(bad, dtype=torch.int32, device="cuda")
    try:
        owq.pack(W, idx)
        print("PACK ACCEPTED", bad, flush=True)
    except owq.OwqError as e:
        print("PACK STATUS", e.status, flush=True)
    p2 = dict(p, weak_idx=idx)
    try:
        owq.linear(p2, x)
        print("LINEAR ACCEPTED", bad, flush=True)
    except owq.OwqError as e:
        print("LINEAR STATUS", e.status, flush=True)
torch.cuda.synchronize()
"""


def test_owq_check_rejects_bad_weak_indices():
    env = dict(os.environ, OWQ_CHECK="1")
    r = subprocess.run([sys.executable, "-c", CHILD], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = r.stdout.splitlines()
    assert "GOOD OK" in lines
    assert lines.count("PACK STATUS 3") == 4, r.stdout
    assert lines.count("LINEAR STATUS 3") == 4, r.stdout
