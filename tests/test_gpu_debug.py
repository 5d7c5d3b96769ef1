"""BSATTN_DEBUG=2 on the real kernels: every compute call synchronises its stream,
checks for a kernel failure and for writes past the workspace bytes it needs (a
canary after them), and logs calls and launches.  Run in a child process, since
the level is read once per process."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import torch
from block_sparse_long_bsattn_amd import _lib as B
from block_sparse_long_bsattn_amd import inputs as I
shape = (2, 2, 1024, 64)
q, k, v, do = (torch.from_numpy(I.make_tensor(s, shape, "bf16")[0].view("int16")).view(torch.bfloat16).cuda()
               for s in (I.SEED_Q, I.SEED_K, I.SEED_V, I.SEED_DO))
h = B.bsattn_layout_build(1024, 64, 2, [0, 15], 3, 3, 5)
o, olo = torch.empty_like(q), torch.empty_like(q)
lse = torch.empty((2, 2, 1024), dtype=torch.float32, device="cuda")
wsf = torch.empty(B.bsattn_fwd_workspace(h, 2) + 64, dtype=torch.uint8, device="cuda")
wsb = torch.empty(B.bsattn_bwd_workspace(h, 2) + 64, dtype=torch.uint8, device="cuda")
B.bsattn_fwd(h, q, k, v, o, lse, wsf, o_lo=olo)
dq, dk, dv = (torch.empty_like(q) for _ in range(3))
B.bsattn_bwd(h, q, k, v, o, lse, do, dq, dk, dv, wsb, o_lo=olo)
torch.cuda.synchronize()
B.bsattn_layout_destroy(h)
print("ok", flush=True)
'''


def test_debug_level2_on_the_gpu():
    env = dict(os.environ, BSATTN_DEBUG="2", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", CHILD], env=env, capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-3000:]
    for line in ("[bsattn] call fwd", "[bsattn] launch bs_fwd_bf16", "[bsattn] done fwd",
                 "[bsattn] launch bs_bwd_dkdv", "[bsattn] done bwd"):
        assert line in r.stderr, (line, r.stderr[-3000:])
    assert "[bsattn] error" not in r.stderr
