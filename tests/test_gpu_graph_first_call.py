"""A forward + backward captured into a HIP graph as the very first library
calls of a process (the library has created no stream or event yet): the
replays equal the eager results bit for bit. Runs in a fresh child process,
since this test process has called the library before."""
import os
import subprocess
import sys

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
import gated_delta_rule_74_amd as gdn
import gdn_inputs as gi

x = gi.gen_seq(1, 2048, 4, 56, 56, "bf16", seed=7840, h0="randn", with_do=True, decay="weak")
def d(a):
    if isinstance(a, gi.Tensor):
        return torch.from_numpy(a.data.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()
q, k, v, g, beta, A_log, h0, do = (d(x[n]) for n in ("q", "k", "v", "g", "beta", "A_log", "h0", "do"))
o = torch.empty_like(v)
hT = torch.empty_like(h0)
ctx = torch.empty(gdn.context_size(q, v), dtype=torch.uint8, device="cuda")
fws = torch.empty(gdn.fwd_workspace_size(q, v), dtype=torch.uint8, device="cuda")
bws = torch.empty(gdn.bwd_workspace_size(q, v), dtype=torch.uint8, device="cuda")
grads = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
         "dg": torch.empty_like(g), "dbeta": torch.empty_like(beta), "dA_log": torch.empty_like(A_log),
         "dh0": torch.empty_like(h0)}
def step():
    gdn.fwd(q, k, v, g, beta, A_log, h0, o=o, hT=hT, context=ctx, workspace=fws)
    gdn.bwd(q, k, v, g, beta, A_log, do, h0, None, context=ctx, workspace=bws, out=grads)
torch.cuda.synchronize()
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):
    step()                      # first library calls of this process
outs = {"o": o, "hT": hT, **{n: t for n, t in grads.items() if t is not None}}
got = []
for rep in range(3):
    for t in outs.values():
        t.zero_()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    got.append({n: t.clone() for n, t in outs.items()})
step()                          # eager, now with the second stream available
torch.cuda.synchronize()
for rep, r in enumerate(got):
    for n, t in outs.items():
        assert torch.equal(r[n], t), f"{n} differs on replay {rep}"
print("first-call capture: 3 replays equal the eager pass", flush=True)
"""


def test_first_library_call_captured():
    say("graph capture of the first library calls (child process)")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, timeout=300)
    print(r.stdout[-2000:], r.stderr[-4000:], flush=True)
    assert r.returncode == 0, f"child exited with {r.returncode}"
    assert "3 replays equal" in r.stdout
